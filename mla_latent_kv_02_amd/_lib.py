"""ctypes declarations of libmla's C ABI (include/libmla.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
import re
from ctypes import POINTER, c_float, c_int32, c_int64, c_size_t, c_void_p, c_char_p

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmla.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "libmla.h")

MLA_OK, MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE, MLA_ERR_HIP = 0, 1, 2, 3, 4
MLA_F32, MLA_BF16 = 0, 1
MLA_FMT_F32, MLA_FMT_BF16, MLA_FMT_INT4, MLA_FMT_INT2 = 0, 1, 2, 3
MLA_DEQUANT_PARTITION, MLA_DEQUANT_ROWS = 0, 1
DEQUANT_FAMILY = {"partition": MLA_DEQUANT_PARTITION, "rows": MLA_DEQUANT_ROWS}
FMT_BY_NAME = {"f32": MLA_FMT_F32, "bf16": MLA_FMT_BF16, "int4": MLA_FMT_INT4, "int2": MLA_FMT_INT2}


class CacheDesc(ctypes.Structure):
    _fields_ = [("d_c", c_int32), ("d_r", c_int32), ("block_size", c_int32), ("latent_fmt", c_int32),
                ("rope_fmt", c_int32), ("latent_group", c_int32), ("rope_group", c_int32)]


class DecodeArgs(ctypes.Structure):
    _fields_ = [("q_lat", c_void_p), ("q_rope", c_void_p), ("q_dtype", c_int32), ("cache_pool", c_void_p),
                ("num_blocks", c_int64), ("cache", CacheDesc), ("block_table", c_void_p),
                ("block_table_stride", c_int32), ("seq_lens", c_void_p), ("max_seq_len", c_int32), ("total_seq_len", c_int64),
                ("batch", c_int32), ("s_q", c_int32), ("num_heads", c_int32), ("sm_scale", c_float),
                ("num_splits", c_int32), ("o_lat", c_void_p), ("o_dtype", c_int32), ("lse", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


class GqaArgs(ctypes.Structure):
    _fields_ = [("q_nope", c_void_p), ("q_rope", c_void_p), ("cache_pool", c_void_p), ("num_blocks", c_int64),
                ("num_groups", c_int32), ("d_n", c_int32), ("d_v", c_int32), ("d_r", c_int32),
                ("block_table", c_void_p), ("block_table_stride", c_int32), ("seq_lens", c_void_p),
                ("max_seq_len", c_int32), ("total_seq_len", c_int64), ("batch", c_int32), ("s_q", c_int32),
                ("num_heads", c_int32), ("sm_scale", c_float), ("num_splits", c_int32), ("out", c_void_p),
                ("lse", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t)]


_SIGS = {
    "mla_abi_version": (c_int32, []),
    "mla_status_string": (c_char_p, [c_int32]),
    "mla_cache_block_bytes": (c_int64, [POINTER(CacheDesc)]),
    "mla_cache_plane_offsets": (c_int32, [POINTER(CacheDesc), POINTER(c_int64)]),
    "mla_absorb_q": (c_int32, [c_void_p, c_int64, c_int64, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                               c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "mla_out_proj": (c_int32, [c_void_p, c_int64, c_int64, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                               c_int32, c_int32, c_int32, c_int32, c_void_p]),
    "mla_decode_workspace_size": (c_int32, [POINTER(DecodeArgs), POINTER(c_size_t)]),
    "mla_decode_workspace_size_for": (c_int32, [POINTER(DecodeArgs), c_int32, POINTER(c_size_t)]),
    "mla_decode_plan": (c_int32, [POINTER(DecodeArgs), c_int32, POINTER(c_int32), POINTER(c_int32)]),
    "mla_decode_paged": (c_int32, [POINTER(DecodeArgs), c_void_p]),
    "mla_decode_paged_noalloc": (c_int32, [POINTER(DecodeArgs), c_void_p]),
    "mla_decode_mixed": (c_int32, [POINTER(DecodeArgs), POINTER(DecodeArgs), POINTER(DecodeArgs), c_void_p, c_int32,
                                   c_void_p, c_void_p, c_size_t, c_void_p]),
    "mla_decode_mixed_workspace_size": (c_int32, [POINTER(DecodeArgs), POINTER(DecodeArgs), POINTER(DecodeArgs),
                                                  POINTER(c_size_t)]),
    "mla_dequant_blocks": (c_int32, [c_void_p, c_int64, POINTER(CacheDesc), c_void_p, c_int32, c_int32,
                                     c_void_p, c_void_p]),
    "mla_append_kv": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_int32, c_void_p, c_int64, c_void_p,
                                c_int64, POINTER(CacheDesc), c_void_p]),
    "mla_gqa_block_bytes": (c_int64, [c_int32, c_int32, c_int32, c_int32]),
    "mla_gqa_expand": (c_int32, [c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, c_void_p, c_int64, c_void_p, c_int64, c_void_p]),
    "mla_gqa_workspace_size": (c_int32, [POINTER(GqaArgs), POINTER(c_size_t)]),
    "mla_gqa_decode_paged": (c_int32, [POINTER(GqaArgs), c_void_p]),
    "mla_hadamard_rotate": (c_int32, [c_void_p, c_int32, c_int32, c_int64, c_int64, c_int64, c_int64, c_int64,
                                      c_void_p]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree libmla.so; raise if it has not been built (there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libmla.so not found at {LIB_PATH}; build it with "
                          "`python -m mla_latent_kv_02_amd.build` (no CPU fallback exists)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def header_functions():
    """Names of the functions include/libmla.h declares."""
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", src)))
