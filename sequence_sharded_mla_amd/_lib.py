"""ctypes declarations of libmla_dcp.so (mirrors include/mla_dcp.h).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla_dcp.so")

MLA_OK = 0
MLA_ERR_NULL = 1
MLA_ERR_SHAPE = 2
MLA_ERR_SHARD = 3
MLA_ERR_UNSUPPORTED = 4
MLA_ERR_WORKSPACE = 5
MLA_ERR_DEVICE = 6
MLA_ERR_ALIGN = 7

MLA_F32 = 0
MLA_BF16 = 1
MLA_FP8_DS = 2

MLA_DEVERR_BLOCK_TABLE = 1
MLA_DEVERR_INDEX = 2
MLA_DEVERR_SLOT = 4
MLA_DEVERR_SCORES = 8
MLA_DEVERR_QUERY = 16


class MLADecodeDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("q_len", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("rope_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks", ctypes.c_int32),
        ("topk", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("pool_blocks", ctypes.c_int64),
    ]


_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_pdesc = ctypes.POINTER(MLADecodeDesc)

# name -> (restype, argtypes); keep in the order of the header
SIGNATURES = {
    "mla_status_string": (ctypes.c_char_p, [_i32]),
    "mla_shard_local_len": (_i32, [_i32, _i32, _i32]),
    "mla_kv_row_bytes": (_i64, [_i32]),
    "mla_decode_workspace_size": (_i32, [_pdesc, _i32, ctypes.POINTER(_i64)]),
    "mla_decode_partial": (_i32, [_pdesc, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                  _i64, _vp]),
    "mla_decode_partial_noalloc": (_i32, [_pdesc, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp,
                                          _vp]),
    "mla_decode_partial_shards": (_i32, [_pdesc, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _vp,
                                         _vp, _vp, _i64, _vp]),
    "mla_decode_partial_shards_varlen": (_i32, [_pdesc, _vp, _vp, _vp, _vp, _vp, _i32, _vp, _i32, _i32,
                                                _i32, _vp, _vp, _vp, _i64, _vp]),
    "mla_lse_merge": (_i32, [_i32, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp]),
    "mla_localize_indices": (_i32, [_vp, _i64, _i32, _i32, _vp, _vp]),
    "mla_dcp_slot_mapping": (_i32, [_vp, _vp, _i64, _vp, _i32, _i32, _i64, _i32, _i32, _i32, _vp,
                                    _vp, _vp]),
    "mla_kv_write": (_i32, [_vp, _i32, _i64, _vp, _i32, _vp, _i64, _vp, _vp]),
    "mla_dcp_kv_write": (_i32, [_vp, _i32, _vp, _vp, _i64, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                                _vp, _i64, _vp, _vp]),
    "mla_topk_local": (_i32, [_vp, _i64, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp]),
    "mla_topk_local_varlen": (_i32, [_vp, _i64, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp,
                                     _vp, _vp]),
    "mla_topk_merge": (_i32, [_vp, _vp, _i32, _i64, _i32, _i32, _vp, _vp]),
    "mla_get_device_error": (_i32, [_vp, ctypes.POINTER(_i32), _vp]),
    "mla_clear_device_error": (_i32, [_vp, _vp]),
}

_lib = None


def load():
    """Load the shared library (once) and declare every entry point."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first "
            "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
