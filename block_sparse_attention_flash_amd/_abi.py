"""ctypes view of include/bsattn.h (structures and prototypes only)."""

from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "lib", "libbsattn.so")

BSATTN_OK = 0
BSATTN_ERR_INVALID_ARG = 1
BSATTN_ERR_UNSUPPORTED = 2
BSATTN_ERR_CAPACITY = 3
BSATTN_ERR_HIP = 4

BSATTN_BF16 = 0
BSATTN_FP32 = 1

# every symbol declared in include/bsattn.h
EXPORTED = (
    "bsattn_status_string", "bsattn_last_error", "bsattn_version",
    "bsattn_build_block_index", "bsattn_validate_block_index", "bsattn_tile_order_lpt",
    "bsattn_build_schedule", "bsattn_schedule_tile_order", "bsattn_prefill_group_major",
    "bsattn_prefill_workspace_size", "bsattn_prefill_fwd",
    "bsattn_transpose_block_index", "bsattn_prefill_bwd_workspace_size", "bsattn_prefill_bwd",
    "bsattn_build_dkdv_schedule",
    "bsattn_block_index_from_matrix", "bsattn_block_index_from_bitmap", "bsattn_block_index_from_coo",
    "bsattn_decode_workspace_size", "bsattn_decode_num_splits", "bsattn_decode_split_blocks",
    "bsattn_decode_fwd", "bsattn_decode_check", "bsattn_decode_fwd_noalloc",
    "bsattn_calibrate_threshold",
)


class Segment(C.Structure):
    _fields_ = [("kind", C.c_int32), ("start", C.c_int32), ("len", C.c_int32), ("frames", C.c_int32),
                ("grid_h", C.c_int32), ("grid_w", C.c_int32), ("radius", C.c_int32), ("t_radius", C.c_int32),
                ("unit", C.c_int32)]


class MaskSpec(C.Structure):
    _fields_ = [("n_valid", C.c_int32), ("n_segments", C.c_int32), ("segments", C.POINTER(Segment)),
                ("anchor_start", C.c_int32), ("anchor_len", C.c_int32)]


class PrefillArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32),
                ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("out", C.c_void_p),
                ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("Nq", C.c_int32), ("Nk", C.c_int32),
                ("d", C.c_int32),
                ("q_stride", C.c_int64 * 3), ("k_stride", C.c_int64 * 3), ("v_stride", C.c_int64 * 3),
                ("o_stride", C.c_int64 * 3),
                ("row_ptr", C.c_void_p), ("col_idx", C.c_void_p), ("tile_order", C.c_void_p),
                ("n_valid", C.c_int32), ("scale", C.c_float), ("lam", C.c_float), ("causal", C.c_int32),
                ("Br", C.c_int32), ("Bc", C.c_int32),
                ("tile_counters", C.c_void_p), ("block_state", C.c_void_p),
                ("row_counters", C.c_void_p),
                ("block_order", C.c_int32),
                ("sched_items", C.c_void_p), ("n_items", C.c_int32), ("sched_merges", C.c_void_p),
                ("n_merges", C.c_int32), ("n_slots", C.c_int32), ("workspace", C.c_void_p),
                ("workspace_bytes", C.c_size_t), ("lse", C.c_void_p)]


class BwdArgs(C.Structure):
    _fields_ = [("dtype", C.c_int32),
                ("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("out", C.c_void_p), ("dout", C.c_void_p),
                ("lse", C.c_void_p), ("dq", C.c_void_p), ("dk", C.c_void_p), ("dv", C.c_void_p),
                ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("Nq", C.c_int32), ("Nk", C.c_int32),
                ("d", C.c_int32),
                ("q_stride", C.c_int64 * 3), ("k_stride", C.c_int64 * 3), ("v_stride", C.c_int64 * 3),
                ("o_stride", C.c_int64 * 3), ("do_stride", C.c_int64 * 3), ("dq_stride", C.c_int64 * 3),
                ("dk_stride", C.c_int64 * 3), ("dv_stride", C.c_int64 * 3),
                ("row_ptr", C.c_void_p), ("col_idx", C.c_void_p), ("col_ptr", C.c_void_p), ("row_idx", C.c_void_p),
                ("n_valid", C.c_int32), ("scale", C.c_float), ("causal", C.c_int32), ("Br", C.c_int32),
                ("Bc", C.c_int32), ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("block_state", C.c_void_p),
                ("dq_items", C.c_void_p), ("dq_n_items", C.c_int32), ("dq_merges", C.c_void_p),
                ("dq_n_merges", C.c_int32), ("dq_n_slots", C.c_int32),
                ("kv_items", C.c_void_p), ("kv_n_items", C.c_int32), ("kv_merges", C.c_void_p),
                ("kv_n_merges", C.c_int32), ("kv_n_slots", C.c_int32)]


class DecodeArgs(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k_cache", C.c_void_p), ("v_cache", C.c_void_p), ("out", C.c_void_p),
                ("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("L", C.c_int32), ("Lmax", C.c_int32),
                ("d", C.c_int32),
                ("q_stride", C.c_int64 * 2), ("kv_stride", C.c_int64 * 3), ("o_stride", C.c_int64 * 2),
                ("scale", C.c_float), ("lam", C.c_float), ("Bc", C.c_int32), ("num_splits", C.c_int32),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("counters", C.c_void_p), ("block_state", C.c_void_p), ("block_order", C.c_int32),
                ("max_scope", C.c_int32), ("decisions", C.c_int32)]


def load(path: str = None) -> C.CDLL:
    """Load libbsattn.so (``BSATTN_LIB`` overrides the in-tree path)."""
    path = path or os.environ.get("BSATTN_LIB") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_attention_flash_amd.build` "
            "(there is no fallback implementation)")
    lib = C.CDLL(path)
    lib.bsattn_status_string.restype = C.c_char_p
    lib.bsattn_status_string.argtypes = [C.c_int]
    lib.bsattn_last_error.restype = C.c_char_p
    lib.bsattn_last_error.argtypes = []
    lib.bsattn_version.restype = C.c_int
    lib.bsattn_build_block_index.restype = C.c_int
    lib.bsattn_build_block_index.argtypes = [C.POINTER(MaskSpec), C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                             C.c_void_p, C.c_void_p, C.c_int64, C.POINTER(C.c_int64)]
    lib.bsattn_validate_block_index.restype = C.c_int
    lib.bsattn_validate_block_index.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32]
    lib.bsattn_tile_order_lpt.restype = C.c_int
    lib.bsattn_tile_order_lpt.argtypes = [C.c_void_p, C.c_int32, C.c_void_p]
    lib.bsattn_build_schedule.restype = C.c_int
    lib.bsattn_build_schedule.argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                                          C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                                          C.POINTER(C.c_int32)]
    lib.bsattn_schedule_tile_order.restype = C.c_int
    lib.bsattn_schedule_tile_order.argtypes = [C.c_void_p, C.c_int32]
    lib.bsattn_prefill_group_major.restype = C.c_int32
    lib.bsattn_prefill_group_major.argtypes = [C.c_int32] * 5
    lib.bsattn_prefill_workspace_size.restype = C.c_size_t
    lib.bsattn_prefill_workspace_size.argtypes = [C.c_int32] * 4
    lib.bsattn_prefill_fwd.restype = C.c_int
    lib.bsattn_prefill_fwd.argtypes = [C.POINTER(PrefillArgs), C.c_void_p]
    for fn in ("bsattn_block_index_from_matrix", "bsattn_block_index_from_bitmap"):
        getattr(lib, fn).restype = C.c_int
        getattr(lib, fn).argtypes = [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_int64,
                                     C.POINTER(C.c_int64)]
    lib.bsattn_block_index_from_coo.restype = C.c_int
    lib.bsattn_block_index_from_coo.argtypes = [C.c_void_p, C.c_void_p, C.c_int64, C.c_int32, C.c_int32, C.c_void_p,
                                                C.c_void_p, C.c_int64, C.POINTER(C.c_int64)]
    lib.bsattn_transpose_block_index.restype = C.c_int
    lib.bsattn_transpose_block_index.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p,
                                                 C.c_void_p]
    lib.bsattn_prefill_bwd_workspace_size.restype = C.c_size_t
    lib.bsattn_prefill_bwd_workspace_size.argtypes = [C.c_int32] * 7
    lib.bsattn_build_dkdv_schedule.restype = C.c_int
    lib.bsattn_build_dkdv_schedule.argtypes = [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_int32,
                                               C.c_void_p, C.c_int32, C.c_void_p, C.c_int32,
                                               C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.POINTER(C.c_int32)]
    lib.bsattn_prefill_bwd.restype = C.c_int
    lib.bsattn_prefill_bwd.argtypes = [C.POINTER(BwdArgs), C.c_void_p]
    lib.bsattn_decode_workspace_size.restype = C.c_size_t
    lib.bsattn_decode_workspace_size.argtypes = [C.c_int32] * 7
    lib.bsattn_decode_num_splits.restype = C.c_int32
    lib.bsattn_decode_num_splits.argtypes = [C.c_int32] * 7
    lib.bsattn_decode_split_blocks.restype = C.c_int32
    lib.bsattn_decode_split_blocks.argtypes = [C.c_int32] * 7
    lib.bsattn_decode_fwd.restype = C.c_int
    lib.bsattn_decode_fwd.argtypes = [C.POINTER(DecodeArgs), C.c_void_p]
    lib.bsattn_decode_fwd_noalloc.restype = C.c_int
    lib.bsattn_decode_fwd_noalloc.argtypes = [C.POINTER(DecodeArgs), C.c_void_p]
    lib.bsattn_decode_check.restype = C.c_int
    lib.bsattn_decode_check.argtypes = [C.c_void_p, C.POINTER(C.c_int32)]
    lib.bsattn_calibrate_threshold.restype = C.c_int
    lib.bsattn_calibrate_threshold.argtypes = [C.c_double, C.c_void_p, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p,
                                               C.c_double, C.POINTER(C.c_double), C.POINTER(C.c_int32)]
    return lib
