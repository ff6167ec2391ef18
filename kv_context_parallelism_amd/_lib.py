"""ctypes view of libcpattn.so (declarations mirror include/cpattn.h)."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libcpattn.so")

CP_OK, CP_E_INVALID, CP_E_UNSUPPORTED, CP_E_WORKSPACE, CP_E_HIP = range(5)
CP_F32, CP_BF16, CP_FP8_E4M3FN = range(3)
CP_SLOT_NOT_MINE, CP_SLOT_INVALID = -1, -2
CP_KV_DENSE, CP_KV_PAGED, CP_KV_PAGED_CAUSAL = 0, 1, 2
CP_OP_DECODE_GQA, CP_OP_DECODE_MLA, CP_OP_PREFILL, CP_OP_DECODE_GQA_MTP = 1, 2, 3, 4
CP_MAX_SHARDS = 16

_vp, _i32, _i64, _f32, _int = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                               ctypes.c_int)


class CpGqaArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("k_cache", _vp), ("v_cache", _vp), ("block_table", _vp),
                ("local_len", _vp), ("B", _i32), ("Hq", _i32), ("Hkv", _i32), ("D", _i32),
                ("bs", _i32), ("bt_stride", _i32), ("num_blocks", _i64), ("scale", _f32),
                ("dt", _int), ("out", _vp), ("lse", _vp)]


class CpGqaMtpArgs(ctypes.Structure):
    _fields_ = [("base", CpGqaArgs), ("q_len", _i32), ("dcp_rank", _i32), ("dcp_size", _i32),
                ("interleave", _i32), ("seq_len", _vp)]


class CpMlaArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("kv_cache", _vp), ("block_table", _vp), ("local_len", _vp),
                ("B", _i32), ("H", _i32), ("Dk", _i32), ("Dv", _i32), ("bs", _i32),
                ("bt_stride", _i32), ("num_blocks", _i64), ("scale", _f32), ("kv_dt", _int),
                ("kv_scale", _f32), ("out", _vp), ("lse", _vp)]


class CpPrefillArgs(ctypes.Structure):
    _fields_ = [("q", _vp), ("C", _i32), ("P", _i32), ("pcp_rank", _i32), ("pcp_size", _i32),
                ("Hq", _i32), ("Hkv", _i32), ("D", _i32), ("scale", _f32), ("kv_source", _i32),
                ("k", _vp), ("v", _vp), ("k_cache", _vp), ("v_cache", _vp),
                ("block_table", _vp), ("local_len", _i32), ("bs", _i32), ("bt_stride", _i32),
                ("num_blocks", _i64), ("out", _vp), ("lse", _vp), ("dcp_rank", _i32),
                ("dcp_size", _i32), ("dcp_interleave", _i32)]



class CpKvGatherArgs(ctypes.Structure):
    _fields_ = [("N", _i32), ("I", _i32), ("bs", _i32), ("B", _i32), ("Hkv", _i32), ("D", _i32),
                ("dt", _int), ("k_caches", _vp), ("v_caches", _vp), ("block_tables", _vp),
                ("num_blocks", _vp), ("bt_stride", _i32), ("t0", _i32), ("W", _i32),
                ("seq_len", _vp), ("k_out", _vp), ("v_out", _vp)]

# name -> (restype, argtypes); every function the header declares
SIGNATURES = {
    "cp_status_str": (ctypes.c_char_p, [_int]),
    "cp_last_error": (ctypes.c_char_p, []),
    "cp_abi_version": (_int, []),
    "cp_local_seq_lens": (_int, [_i32, _vp, _i32, _i32, _i32, _vp, _vp]),
    "cp_slot_map": (_int, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _vp,
                           _vp]),
    "cp_cache_write": (_int, [_i64, _vp, _vp, _vp, _i32, _i32, _int, _vp, _vp, _i64, _i32, _vp]),
    "cp_slot_map_cache_write": (_int, [_i32, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                       _i32, _vp, _vp, _vp, _i32, _i32, _int, _vp, _vp, _i64,
                                       _vp]),
    "cp_decode_attn_partial_gqa": (_int, [ctypes.POINTER(CpGqaArgs), _vp, ctypes.c_size_t, _vp]),
    "cp_decode_attn_partial_gqa_noalloc": (_int, [ctypes.POINTER(CpGqaArgs), _vp]),
    "cp_noalloc_scratch_bytes": (ctypes.c_size_t, []),
    "cp_decode_attn_partial_gqa_mtp": (_int, [ctypes.POINTER(CpGqaMtpArgs), _vp, ctypes.c_size_t,
                                              _vp]),
    "cp_decode_attn_partial_mla": (_int, [ctypes.POINTER(CpMlaArgs), _vp, ctypes.c_size_t, _vp]),
    "cp_lse_merge": (_int, [_i32, _i64, _i32, _vp, _vp, _vp, _int, _vp, _vp]),
    "cp_lse_correct": (_int, [_i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "cp_a2a_pack": (_int, [_i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "cp_lse_merge_packed": (_int, [_i32, _i64, _i32, _vp, _i64, _vp, _int, _vp, _vp]),
    "pcp_prefill_attn_causal": (_int, [ctypes.POINTER(CpPrefillArgs), _vp, ctypes.c_size_t, _vp]),
    "cp_kv_gather": (_int, [ctypes.POINTER(CpKvGatherArgs), _vp]),
    "cp_workspace_bytes": (ctypes.c_size_t, [_int, _vp]),
}

_lib = None


def load():
    """Load the built library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m kv_context_parallelism_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if lib.cp_abi_version() != 1:
        raise ImportError("libcpattn ABI version mismatch")
    _lib = lib
    return lib
