"""ctypes declarations of the C ABI in include/fi.h (libfi.so in this folder)."""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
# FI_LIB_PATH selects another build of the same library (the CPU tests run the
# ABI tests once more against a build whose host code carries AddressSanitizer
# and UBSan checks).
LIB_PATH = os.environ.get("FI_LIB_PATH") or os.path.join(HERE, "libfi.so")

FI_OK, FI_ERR_INVALID_ARG, FI_ERR_UNSUPPORTED, FI_ERR_WORKSPACE, FI_ERR_PLAN_MISMATCH, \
    FI_ERR_HIP = range(6)
FI_KIND_DECODE, FI_KIND_APPEND, FI_KIND_CASCADE, FI_KIND_BLOCK_SPARSE = range(4)
FI_DTYPE_BF16, FI_DTYPE_F32 = 0, 1
FI_ENGINE_DEFAULT, FI_ENGINE_MFMA, FI_ENGINE_VALU = range(3)
FI_LAUNCH_DEFAULT, FI_LAUNCH_POD, FI_LAUNCH_SEPARATE = range(3)
FI_KV_BF16, FI_KV_FP8, FI_KV_MXFP4 = range(3)
FI_MERGE_DEFAULT, FI_MERGE_FUSED, FI_MERGE_SEPARATE = range(3)
FI_KV_LAYOUT_PAGED, FI_KV_LAYOUT_RAGGED = range(2)
FI_ITEM_INTS, FI_MERGE_INTS = 12, 6
FI_NOALLOC_SCRATCH_BYTES = 16 << 20

STATUS_NAMES = {0: "FI_OK", 1: "FI_ERR_INVALID_ARG", 2: "FI_ERR_UNSUPPORTED",
                3: "FI_ERR_WORKSPACE", 4: "FI_ERR_PLAN_MISMATCH", 5: "FI_ERR_HIP"}


class PlanDesc(ctypes.Structure):
    _fields_ = [(n, c_int32) for n in (
        "kind", "batch", "num_qo_heads", "num_kv_heads", "head_dim", "page_size", "causal",
        "deterministic", "det_chunk_pages", "min_chunk_pages", "num_cus", "workers_per_cu",
        "num_prefix_groups", "decode_engine", "max_prefix_depth", "launch", "pod_wide_blocks", "cap_batch", "cap_kv_pages",
        "cap_qo_tokens", "cap_prefix_pages", "kv_format", "merge_mode", "kv_layout")]


I32P = POINTER(c_int32)


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("kind", c_int32), ("num_levels", c_int32), ("num_workers", c_int32 * 2),
        ("min_chunk_pages", c_int32 * 2), ("rows_per_block", c_int32 * 2), ("chunk_pages", c_int32 * 2),
        ("num_items", c_int32 * 2), ("items", I32P * 2), ("worker_indptr", I32P * 2),
        ("num_merges", c_int32), ("merges", I32P), ("num_parts", c_int32), ("parts", I32P),
        ("num_qlist", c_int32), ("qlist", I32P), ("num_part_rows", c_int32),
        ("num_scatter", c_int32), ("dev_bytes_used", c_size_t), ("host_bytes_used", c_size_t),
        ("pod_wide_blocks", c_int32), ("num_plist", c_int32), ("plist", I32P),
        ("fused_merge", c_int32), ("item_rec", I32P), ("num_empty_recs", c_int32),
        ("empty_recs", I32P), ("wg_fold", c_int32),
    ]


# name -> (restype, argtypes); exactly the functions include/fi.h declares
SIGNATURES = {
    "fi_workspace_size": (c_int32, [POINTER(PlanDesc), c_int64, c_int64, c_int64,
                                    POINTER(c_size_t), POINTER(c_size_t)]),
    "fi_plan": (c_int32, [POINTER(PlanDesc), I32P, I32P, I32P, I32P, I32P, I32P, I32P, c_void_p,
                          c_size_t, c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    "fi_plan_destroy": (None, [c_void_p]),
    "fi_plan_get_info": (c_int32, [c_void_p, POINTER(PlanInfo)]),
    "fi_paged_decode": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                  c_void_p, c_void_p, c_void_p]),
    "fi_paged_decode_fp8": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                      c_void_p]),
    "fi_paged_decode_mxfp4": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_float, c_void_p, c_void_p,
                                        c_void_p]),
    "fi_paged_decode_noalloc": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_float, c_void_p, c_void_p, c_void_p]),
    "fi_check_page_tables": (c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_void_p,
                                       c_void_p]),
    "fi_paged_append": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                  c_void_p, c_float, c_void_p, c_void_p, c_void_p]),
    "fi_cascade": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                             c_float, c_void_p, c_void_p, c_void_p]),
    "fi_workspace_size_block_sparse": (c_int32, [POINTER(PlanDesc), c_int32, c_int32, c_int32,
                                                 c_int32, POINTER(c_size_t),
                                                 POINTER(c_size_t)]),
    "fi_plan_block_sparse": (c_int32, [POINTER(PlanDesc), c_int32, c_int32, c_int32, I32P,
                                       c_int32, I32P, c_void_p, I32P, c_void_p, c_size_t,
                                       c_void_p, c_size_t, c_void_p, POINTER(c_void_p)]),
    "fi_workspace_size_block_sparse_batch": (c_int32, [POINTER(PlanDesc), c_int32, I32P, I32P,
                                                       I32P, I32P, POINTER(c_size_t),
                                                       POINTER(c_size_t)]),
    "fi_plan_block_sparse_batch": (c_int32, [POINTER(PlanDesc), c_int32, I32P, I32P, I32P, I32P,
                                             I32P, I32P, c_void_p, I32P, I32P, c_void_p,
                                             c_size_t, c_void_p, c_size_t, c_void_p,
                                             POINTER(c_void_p)]),
    "fi_block_sparse_attention": (c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_float,
                                            c_void_p, c_void_p, c_void_p]),
    "fi_merge_states": (c_int32, [c_void_p, c_int32, c_void_p, c_int32, c_int32, c_int32,
                                  c_int32, c_void_p, c_int32, c_void_p, c_void_p]),
    "fi_last_error": (c_char_p, []),
    "fi_timer_begin": (c_int32, [c_int32]),
    "fi_timer_end": (c_int32, [POINTER(c_double), POINTER(c_int32)]),
}

_lib = None


def load():
    """Load libfi.so (raises if it was not built: there is no fallback path)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it first (python -m paged_kv_attention_amd.build "
                "or __graft_entry__.build()); there is no non-HIP fallback")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


class FIError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().fi_last_error().decode(errors="replace")
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


def check(status: int, where: str) -> None:
    if status != FI_OK:
        raise FIError(status, where)
